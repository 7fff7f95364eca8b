// Reduction and fan-out kernels for gfx950 (CDNA4, wave64).
//
// Every collective is a list of jobs; a job is one ring segment c of one
// tensor.  A job either folds R inputs element by element, in the rank order
// (c+1), (c+2), ..., c that a ring reduce-scatter leaves at segment c's owner
// (ruCCL README (ja), "CUDA tensor example": ring AllReduce over logical ranks
// on one GPU), or copies one input bit for bit (broadcast, all-gather, the
// ring's all-gather phase).  The result is written to a set of ranks' outputs.
//
// The work is HBM streaming with no reuse: 16-byte vector loads and stores per
// lane, R loads in flight per vector, non-temporal hints by default.  A job's
// elements split into a scalar head (until every pointer of the job is 16-byte
// aligned), a body of 16-byte vectors, and a scalar tail (fewer than 4
// elements); head and tail are done by the lanes of the job's first tile.
// Jobs whose pointers disagree modulo 16 bytes run element by element.
// Each element is read and written by exactly one lane, and there are no
// atomics, so the summation order is the documented one whatever the grid.
#include <hip/hip_runtime.h>

#include "rc_internal.h"

namespace rc {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

// ---------------------------------------------------------------- operators
// Each operator works on raw 32-bit patterns.

struct OpSumF32 {
    static constexpr bool kCanMean = true;
    __device__ __forceinline__ static uint32_t apply(uint32_t a, uint32_t b) {
        return as_u(as_f(a) + as_f(b));
    }
    __device__ __forceinline__ static u32x4 apply4(u32x4 a, u32x4 b) {
        f32x4 r = __builtin_bit_cast(f32x4, a) + __builtin_bit_cast(f32x4, b);
        return __builtin_bit_cast(u32x4, r);
    }
};

struct OpSumI32 {  // two's-complement wrap: unsigned add
    static constexpr bool kCanMean = false;
    __device__ __forceinline__ static uint32_t apply(uint32_t a, uint32_t b) { return a + b; }
    __device__ __forceinline__ static u32x4 apply4(u32x4 a, u32x4 b) { return a + b; }
};

struct OpMaxI32 {
    static constexpr bool kCanMean = false;
    __device__ __forceinline__ static uint32_t apply(uint32_t a, uint32_t b) {
        int32_t x = (int32_t)a, y = (int32_t)b;
        return (uint32_t)(x > y ? x : y);
    }
    __device__ __forceinline__ static u32x4 apply4(u32x4 a, u32x4 b) {
        u32x4 r;
        r.x = apply(a.x, b.x);
        r.y = apply(a.y, b.y);
        r.z = apply(a.z, b.z);
        r.w = apply(a.w, b.w);
        return r;
    }
};

// float32 max: any NaN gives the quiet NaN 0x7FC00000; equal values keep the
// bitwise AND of their patterns, which picks -0 only when both are -0 and is
// the identity otherwise; else the larger value.  Commutative and associative,
// so the fold order does not change it.
struct OpMaxF32 {
    static constexpr bool kCanMean = false;
    __device__ __forceinline__ static uint32_t apply(uint32_t a, uint32_t b) {
        float x = as_f(a), y = as_f(b);
        if (x != x || y != y) return 0x7FC00000u;
        if (x == y) return a & b;
        return x > y ? a : b;
    }
    __device__ __forceinline__ static u32x4 apply4(u32x4 a, u32x4 b) {
        u32x4 r;
        r.x = apply(a.x, b.x);
        r.y = apply(a.y, b.y);
        r.z = apply(a.z, b.z);
        r.w = apply(a.w, b.w);
        return r;
    }
};

// Mean: one correctly rounded float32 division of the finished fold by R
// (hipcc keeps float division IEEE-exact; for R a power of two the compiler
// may use the exact reciprocal, which gives the same bits).
template <int R>
__device__ __forceinline__ uint32_t mean1(uint32_t acc) {
    return as_u(as_f(acc) / (float)R);
}
template <int R>
__device__ __forceinline__ u32x4 mean4(u32x4 acc) {
    f32x4 r = __builtin_bit_cast(f32x4, acc) / (float)R;
    return __builtin_bit_cast(u32x4, r);
}

// ---------------------------------------------------------------- memory

template <bool NT>
__device__ __forceinline__ u32x4 ld4(const uint32_t* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else return *reinterpret_cast<const u32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ void st4(uint32_t* p, u32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    else *reinterpret_cast<u32x4*>(p) = v;
}
template <bool NT>
__device__ __forceinline__ uint32_t ld1(const uint32_t* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ void st1(uint32_t* p, uint32_t v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// ---------------------------------------------------------------- one job
//
// in[k] is the k-th operand of the fold at the job's first element (the ring
// order of the job's segment); out(o) is rank o's output at that element
// (an Outs).

template <class Op>
__device__ __forceinline__ uint32_t op2(uint32_t a, uint32_t b) { return Op::apply(a, b); }
template <class Op>
__device__ __forceinline__ u32x4 op2(u32x4 a, u32x4 b) { return Op::apply4(a, b); }

// Left fold of the operands in the order given.
template <int NIN, class Op, class V>
__device__ __forceinline__ V fold(const V (&x)[NIN]) {
    V acc = x[0];
#pragma unroll
    for (int k = 1; k < NIN; ++k) acc = op2<Op>(acc, x[k]);
    return acc;
}

// Output pointers of up to NR ranks, all read when the struct is built.  A
// pointer read inside each output's store branch would cost one dependent
// scalar load per output after the data has arrived, and a wave holds its
// slot on the CU all that time.  pin() makes the values live at that point,
// so the loads are issued together and their wait overlaps the HBM loads.
template <int NR>
struct Outs {
    uint32_t* base[NR];
    int64_t off;  // element offset added to every rank's pointer
    __device__ __forceinline__ uint32_t* operator()(int o) const { return base[o] + off; }
    __device__ __forceinline__ void pin() const {
#pragma unroll
        for (int o = 0; o < NR; ++o) asm volatile("" ::"s"(base[o]));
    }
};

template <int NR>
__device__ __forceinline__ Outs<NR> outs_of(void* const* ptrs, int64_t off) {
    Outs<NR> r;
#pragma unroll
    for (int o = 0; o < NR; ++o) r.base[o] = static_cast<uint32_t*>(ptrs[o]);
    r.off = off;
    return r;
}

// With ACC, operand k is acc[k] + in[k] (an accumulator plus the last
// gradient, one add per element with the reduction's Sum), added before the fold.
template <int NIN, int NR, class Op, bool NT, bool ACC, class OutF>
__device__ __forceinline__ void element(const uint32_t* const (&in)[NIN], const uint32_t* const (&ac)[NIN],
                                        int64_t e, const OutF& out, uint32_t mask, bool mean) {
    uint32_t x[NIN];
#pragma unroll
    for (int k = 0; k < NIN; ++k) x[k] = ld1<NT>(in[k] + e);
    if constexpr (ACC) {
        uint32_t y[NIN];
#pragma unroll
        for (int k = 0; k < NIN; ++k) y[k] = ld1<NT>(ac[k] + e);
#pragma unroll
        for (int k = 0; k < NIN; ++k) x[k] = op2<Op>(y[k], x[k]);
    }
    uint32_t acc = fold<NIN, Op>(x);
    if constexpr (Op::kCanMean) {
        if (mean) acc = mean1<NIN>(acc);
    }
#pragma unroll
    for (int o = 0; o < NR; ++o)
        if ((mask >> o) & 1u) st1<NT>(out(o) + e, acc);
}

// The element-by-element path in rounds: J elements per lane, kBlock apart
// (each a coalesced 256-byte run across the wave), all loads issued before
// the folds, so that as many bytes are in flight as in a vector round.
template <int NIN, int NR, class Op, int J, bool NT, bool ACC, class OutF>
__device__ __forceinline__ void element_round(const uint32_t* const (&in)[NIN], const uint32_t* const (&ac)[NIN],
                                              int64_t e, const OutF& out, uint32_t mask, bool mean) {
    constexpr int NA = ACC ? NIN : 1;
    uint32_t x[J][NIN];
    uint32_t y[J][NA];
#pragma unroll
    for (int j = 0; j < J; ++j) {
#pragma unroll
        for (int k = 0; k < NIN; ++k) x[j][k] = ld1<NT>(in[k] + e + j * kBlock);
        if constexpr (ACC) {
#pragma unroll
            for (int k = 0; k < NIN; ++k) y[j][k] = ld1<NT>(ac[k] + e + j * kBlock);
        }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
        if constexpr (ACC) {
#pragma unroll
            for (int k = 0; k < NIN; ++k) x[j][k] = op2<Op>(y[j][k], x[j][k]);
        }
        uint32_t acc = fold<NIN, Op>(x[j]);
        if constexpr (Op::kCanMean) {
            if (mean) acc = mean1<NIN>(acc);
        }
#pragma unroll
        for (int o = 0; o < NR; ++o)
            if ((mask >> o) & 1u) st1<NT>(out(o) + e + j * kBlock, acc);
    }
}

// One round: U vectors per lane.  in[k] + off and out(o) + off are uniform
// (the round's first element); lane vectors sit at 32-bit offsets from there.
// Unless FULL, only the first `nv` vectors of the round exist.
template <int NIN, int NR, class Op, int U, bool NT, bool ACC, bool FULL, class OutF>
__device__ __forceinline__ void vec_round(const uint32_t* const (&in)[NIN], const uint32_t* const (&ac)[NIN],
                                          int64_t off, uint32_t nv, const OutF& out, uint32_t mask,
                                          bool mean) {
    const uint32_t tid = threadIdx.x;
    constexpr int NA = ACC ? NIN : 1;
    u32x4 x[U][NIN];
    u32x4 y[U][NA];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t v = (uint32_t)u * kBlock + tid;
        ok[u] = FULL || v < nv;
        if (ok[u]) {
#pragma unroll
            for (int k = 0; k < NIN; ++k) x[u][k] = ld4<NT>((in[k] + off) + (size_t)(v * kVec));
            if constexpr (ACC) {
#pragma unroll
                for (int k = 0; k < NIN; ++k) y[u][k] = ld4<NT>((ac[k] + off) + (size_t)(v * kVec));
            }
        }
    }
    out.pin();
    u32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (ACC) {
#pragma unroll
            for (int k = 0; k < NIN; ++k) x[u][k] = op2<Op>(y[u][k], x[u][k]);
        }
        acc[u] = fold<NIN, Op>(x[u]);
        if constexpr (Op::kCanMean) {
            if (mean) acc[u] = mean4<NIN>(acc[u]);
        }
    }
#pragma unroll
    for (int o = 0; o < NR; ++o) {
        if (!((mask >> o) & 1u)) continue;
        uint32_t* p = out(o) + off;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t v = (uint32_t)u * kBlock + tid;
            if (FULL || ok[u]) st4<NT>(p + (size_t)(v * kVec), acc[u]);
        }
    }
}

// Tile lt of a job of `len` elements.
template <int NIN, int NR, class Op, int U, bool NT, bool ACC, class OutF>
__device__ __forceinline__ void job_tile(const uint32_t* const (&in)[NIN], const uint32_t* const (&ac)[NIN],
                                         const OutF& out, uint32_t mask, int64_t len, int phase, int64_t lt,
                                         int64_t te, bool mean) {
    const int tid = threadIdx.x;
    if (phase == kScalarOnly) {
        // full rounds of 4U elements per lane (a tile holds a whole number of
        // them), then the last tile's remainder one element per lane at a time
        constexpr int J = 4 * U;
        const int64_t e0 = lt * te;
        const int64_t e1 = e0 + te < len ? e0 + te : len;
        int64_t e = e0;
        for (; e + (int64_t)J * kBlock <= e1; e += (int64_t)J * kBlock)
            element_round<NIN, NR, Op, J, NT, ACC>(in, ac, e + tid, out, mask, mean);
        for (e += tid; e < e1; e += kBlock) element<NIN, NR, Op, NT, ACC>(in, ac, e, out, mask, mean);
        return;
    }
    const int64_t h = phase_head((uint8_t)phase);
    const int64_t head = h < len ? h : len;
    const int64_t nvec = (len - head) / kVec;
    const int64_t tail0 = head + nvec * kVec;
    const int64_t tv = te / kVec;
    // a non-zero lead makes tile 0 the lead vectors alone; tile t >= 1 starts
    // at vector lead + (t-1)*tv, on a kTileAlignBytes boundary
    const int64_t l = phase_lead((uint8_t)phase);
    const int64_t lead = l < nvec ? l : nvec;
    const int64_t shift = lead > 0 ? lead - tv : 0;
    const int64_t v0 = lt * tv + shift > 0 ? lt * tv + shift : 0;
    const int64_t v1 = (lt + 1) * tv + shift < nvec ? (lt + 1) * tv + shift : nvec;
    constexpr int64_t kStep = (int64_t)kBlock * U;
    for (int64_t vb = v0; vb < v1; vb += kStep) {
        const int64_t off = head + vb * kVec;
        if (v1 - vb >= kStep) vec_round<NIN, NR, Op, U, NT, ACC, true>(in, ac, off, 0, out, mask, mean);
        else vec_round<NIN, NR, Op, U, NT, ACC, false>(in, ac, off, (uint32_t)(v1 - vb), out, mask, mean);
    }
    if (lt == 0 && (head > 0 || tail0 < len)) {
        const int64_t nscal = head + (len - tail0);  // at most 3 + 3
        if (tid < nscal) {
            const int64_t e = tid < head ? tid : tail0 + (tid - head);
            element<NIN, NR, Op, NT, ACC>(in, ac, e, out, mask, mean);
        }
    }
}

// ---------------------------------------------------------------- kernels

// Job holding tile t: the number of job boundaries at or below t.  Entries of
// tile_prefix past the last job equal the tile total, which t never reaches.
__device__ __forceinline__ int job_of(const JobArgs& a, int t) {
    int c = 0;
#pragma unroll
    for (int j = 1; j < kMaxRanks; ++j) c += t >= a.tile_prefix[j] ? 1 : 0;
    return c;
}

__device__ __forceinline__ uint32_t out_mask_of(const JobArgs& a, int c) {
    uint32_t mask = a.out_mask;
    if (a.out_mode == kOutOwner) mask = 1u << c;
    else if (a.out_mode == kOutMaskButOwner) mask &= ~(1u << c);
    return mask;
}

// Tile lt of fold job c: input k is rank (c+1+k) mod R at element c*in_stride
// (with ACC, plus that rank's accumulator at the same element).
template <int NIN, class Op, int U, bool NT, bool ACC>
__device__ __forceinline__ void fold_tile(const JobArgs& a, int c, int lt) {
    const int64_t start = (int64_t)c * a.seg;
    const int64_t len = a.n - start < a.seg ? a.n - start : a.seg;
    const int64_t ioff = (int64_t)c * a.in_stride;
    const uint32_t* in[NIN];
    const uint32_t* ac[NIN];
#pragma unroll
    for (int k = 0; k < NIN; ++k) {
        int r = c + 1 + k;  // c < NIN, so r < 2 * NIN
        r = r >= NIN ? r - NIN : r;
        in[k] = static_cast<const uint32_t*>(a.in[r]) + ioff;
        ac[k] = ACC ? static_cast<const uint32_t*>(a.acc[r]) + ioff : nullptr;
    }
    const Outs<NIN> out = outs_of<NIN>(a.out, (int64_t)c * a.out_stride);
    job_tile<NIN, NIN, Op, U, NT, ACC>(in, ac, out, out_mask_of(a, c), len, a.phase[c], lt, a.tile_elems,
                                       a.mean != 0);
}

// Tile lt of copy job c: in[c] at element c*in_stride, copied bit for bit to
// the outputs of up to NR ranks.
template <int NR, int U, bool NT>
__device__ __forceinline__ void copy_tile(const JobArgs& a, int c, int lt) {
    const int64_t start = (int64_t)c * a.seg;
    const int64_t len = a.n - start < a.seg ? a.n - start : a.seg;
    const uint32_t* in[1] = {static_cast<const uint32_t*>(a.in[c]) + (int64_t)c * a.in_stride};
    const uint32_t* none[1] = {nullptr};
    const Outs<NR> out = outs_of<NR>(a.out, (int64_t)c * a.out_stride);
    job_tile<1, NR, OpSumI32, U, NT, false>(in, none, out, out_mask_of(a, c), len, a.phase[c], lt,
                                            a.tile_elems, false);
}

// Whole-tile launches (full_tiles): every job has phase 0 and exactly
// gridDim.x tiles of one round (kBlock*kVec*U elements), so workgroup
// (x, y) = (tile, job) does one full round with no head, lead, tail or
// tile-count logic.  These are kernels of their own: the same round inside
// the general kernel, whose other paths shape its register and scalar-load
// scheduling, measured 2-3% slower on the 8-rank fold.
template <int NIN, class Op, int U, bool NT, bool ACC>
__global__ __launch_bounds__(kBlock) void fold_full_kernel(JobArgs a) {
    const int c = blockIdx.y;
    const int64_t e0 = (int64_t)blockIdx.x * (kBlock * kVec * U);
    const int64_t ioff = (int64_t)c * a.in_stride + e0;
    const uint32_t* in[NIN];
    const uint32_t* ac[NIN];
#pragma unroll
    for (int k = 0; k < NIN; ++k) {
        int r = c + 1 + k;
        r = r >= NIN ? r - NIN : r;
        in[k] = static_cast<const uint32_t*>(a.in[r]) + ioff;
        ac[k] = ACC ? static_cast<const uint32_t*>(a.acc[r]) + ioff : nullptr;
    }
    const Outs<NIN> out = outs_of<NIN>(a.out, (int64_t)c * a.out_stride + e0);
    vec_round<NIN, NIN, Op, U, NT, ACC, true>(in, ac, 0, 0, out, out_mask_of(a, c), a.mean != 0);
}

template <int NR, int U, bool NT>
__global__ __launch_bounds__(kBlock) void copy_full_kernel(JobArgs a) {
    const int c = blockIdx.y;
    const int64_t e0 = (int64_t)blockIdx.x * (kBlock * kVec * U);
    const uint32_t* in[1] = {static_cast<const uint32_t*>(a.in[c]) + (int64_t)c * a.in_stride + e0};
    const uint32_t* none[1] = {nullptr};
    const Outs<NR> out = outs_of<NR>(a.out, (int64_t)c * a.out_stride + e0);
    vec_round<1, NR, OpSumI32, U, NT, false, true>(in, none, 0, 0, out, out_mask_of(a, c), false);
}

// Launch shapes: one-shot launches use a 2-D grid, blockIdx.y = job and
// blockIdx.x = tile of the job (workgroups past a short job's last tile exit);
// persistent launches use a 1-D grid that strides over all tiles.
template <int NIN, class Op, int U, bool NT, bool ACC>
__global__ __launch_bounds__(kBlock) void fold_kernel(JobArgs a) {
    if (a.grid_2d) {
        const int c = blockIdx.y;
        const int lt = blockIdx.x;
        if (lt < a.tile_prefix[c + 1] - a.tile_prefix[c]) fold_tile<NIN, Op, U, NT, ACC>(a, c, lt);
        return;
    }
    for (int t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
        const int c = job_of(a, t);
        fold_tile<NIN, Op, U, NT, ACC>(a, c, t - a.tile_prefix[c]);
    }
}

template <int NR, int U, bool NT>
__global__ __launch_bounds__(kBlock) void copy_kernel(JobArgs a) {
    if (a.grid_2d) {
        const int c = blockIdx.y;
        const int lt = blockIdx.x;
        if (lt < a.tile_prefix[c + 1] - a.tile_prefix[c]) copy_tile<NR, U, NT>(a, c, lt);
        return;
    }
    for (int t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
        const int c = job_of(a, t);
        copy_tile<NR, U, NT>(a, c, t - a.tile_prefix[c]);
    }
}

// Batched all-reduce over a job table in device memory.  A tile's job lies
// between the jobs that hold the first tiles of its group and of the next
// group (group_job); a binary search over that range, usually empty, finds it.
struct BatchArgs {
    const BatchJob* jobs;
    const int32_t* group_job;
    const void* const* ptrs;  // [job][2R], or [job][3R] with ACC: operands, accumulators, outputs
    int64_t total_tiles;
    int64_t ngroups;
    int32_t njobs;
    int32_t tile_elems;
    int32_t mean;
    int32_t grid_2d;  // copies: y = job, x = tile of the job
};

__device__ __forceinline__ int find_job(const BatchArgs& a, int64_t t) {
    const int64_t g = t >> kGroupShift;
    int lo = a.group_job[g];
    int hi = g + 1 < a.ngroups ? a.group_job[g + 1] : a.njobs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.jobs[mid].tile_begin <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <int NIN, class Op, int U, bool NT, bool ACC>
__global__ __launch_bounds__(kBlock) void batch_kernel(BatchArgs a) {
    constexpr int kPtrs = (ACC ? 3 : 2) * NIN;
    constexpr int kOut = (ACC ? 2 : 1) * NIN;
    for (int64_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
        const int j = find_job(a, t);
        const BatchJob jb = a.jobs[j];
        const void* const* tp = a.ptrs + (int64_t)j * kPtrs;
        const uint32_t* in[NIN];
        const uint32_t* ac[NIN];
#pragma unroll
        for (int k = 0; k < NIN; ++k) {
            in[k] = static_cast<const uint32_t*>(tp[k]);
            ac[k] = ACC ? static_cast<const uint32_t*>(tp[NIN + k]) : nullptr;
        }
        const Outs<NIN> out = outs_of<NIN>(const_cast<void* const*>(tp + kOut), 0);
        job_tile<NIN, NIN, Op, U, NT, ACC>(in, ac, out, (1u << NIN) - 1u, jb.len, jb.phase, t - jb.tile_begin,
                                           a.tile_elems, a.mean != 0);
    }
}

// Batched copies over a job table (all_to_all_single, the list form of
// all_gather): job j copies tp[0] to the NR destinations tp[1..NR], bit for bit.
template <int NR, int U, bool NT>
__device__ __forceinline__ void copy_job_tile(const BatchArgs& a, int j, int64_t lt) {
    const BatchJob jb = a.jobs[j];
    const void* const* tp = a.ptrs + (int64_t)j * (1 + NR);
    const uint32_t* in[1] = {static_cast<const uint32_t*>(tp[0])};
    const uint32_t* none[1] = {nullptr};
    const Outs<NR> out = outs_of<NR>(const_cast<void* const*>(tp + 1), 0);
    job_tile<1, NR, OpSumI32, U, NT, false>(in, none, out, (1u << NR) - 1u, jb.len, jb.phase, lt, a.tile_elems,
                                            false);
}

// Tiles of a job of `len` elements with alignment phase `phase` (as planned).
__device__ __forceinline__ int64_t tiles_of(int64_t len, int phase, int64_t te) {
    if (phase == kScalarOnly) return (len + te - 1) / te;
    const int64_t h = phase_head((uint8_t)phase);
    const int64_t head = h < len ? h : len;
    const int64_t nvec = (len - head) / kVec;
    const int64_t l = phase_lead((uint8_t)phase);
    const int64_t lead = l < nvec ? l : nvec;
    const int64_t tv = te / kVec;
    const int64_t t = (lead > 0 ? 1 : 0) + (nvec - lead + tv - 1) / tv;
    return t > 1 ? t : 1;
}

template <int NR, int U, bool NT>
__global__ __launch_bounds__(kBlock) void copy_batch_kernel(BatchArgs a) {
    if (a.grid_2d) {
        const int j = blockIdx.y;
        const BatchJob jb = a.jobs[j];
        if (blockIdx.x < tiles_of(jb.len, jb.phase, a.tile_elems)) copy_job_tile<NR, U, NT>(a, j, blockIdx.x);
        return;
    }
    for (int64_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
        const int j = find_job(a, t);
        copy_job_tile<NR, U, NT>(a, j, t - a.jobs[j].tile_begin);
    }
}

// A copy batch whose table travels in the kernel arguments: job j =
// blockIdx.y copies ptrs[j*(1+NR)] to the next NR pointers; every job has
// len elements.
struct CopyArgs {
    const void* ptrs[kMaxCopyArgPtrs];
    int64_t len;
    int32_t tile_elems;
    int32_t pad;
    uint8_t phase[kMaxCopyArgJobs];
};

template <int NR, int U, bool NT>
__global__ __launch_bounds__(kBlock) void copy_args_kernel(CopyArgs a) {
    const int j = blockIdx.y;
    const int phase = a.phase[j];
    if (blockIdx.x >= tiles_of(a.len, phase, a.tile_elems)) return;
    const void* const* tp = a.ptrs + j * (1 + NR);
    const uint32_t* in[1] = {static_cast<const uint32_t*>(tp[0])};
    const uint32_t* none[1] = {nullptr};
    const Outs<NR> out = outs_of<NR>(const_cast<void* const*>(tp + 1), 0);
    job_tile<1, NR, OpSumI32, U, NT, false>(in, none, out, (1u << NR) - 1u, a.len, phase, blockIdx.x,
                                            a.tile_elems, false);
}

// The whole-tile form of copy_args_kernel (full_tiles): job j = blockIdx.y,
// one full round at element blockIdx.x * kBlock*kVec*U of the job.
template <int NR, int U, bool NT>
__global__ __launch_bounds__(kBlock) void copy_args_full_kernel(CopyArgs a) {
    const void* const* tp = a.ptrs + blockIdx.y * (1 + NR);
    const int64_t e0 = (int64_t)blockIdx.x * (kBlock * kVec * U);
    const uint32_t* in[1] = {static_cast<const uint32_t*>(tp[0]) + e0};
    const uint32_t* none[1] = {nullptr};
    const Outs<NR> out = outs_of<NR>(const_cast<void* const*>(tp + 1), e0);
    vec_round<1, NR, OpSumI32, U, NT, false, true>(in, none, 0, 0, out, 0xFFFFFFFFu >> (32 - NR), false);
}

// ---------------------------------------------------------------- dispatch

// Vectors per lane per round: about eight 16-byte loads in flight per lane,
// counting an accumulator's loads with the operands'.
template <int NIN, bool ACC>
constexpr int kUnroll = unroll_for(ACC ? 2 * NIN : NIN);

using FoldFn = void (*)(JobArgs);
using BatchFn = void (*)(BatchArgs);

// U1: the whole-tile all-reduce of 4-7 ranks with one vector per lane (the
// planner halves its tiles); every other launch uses kUnroll.
template <int NIN, class Op, bool NT, bool ACC, bool FULL, bool U1>
FoldFn fold_ptr() {
    if constexpr (FULL && U1 && NIN >= 4 && NIN < 8 && !ACC) return fold_full_kernel<NIN, Op, 1, NT, ACC>;
    else if constexpr (FULL) return fold_full_kernel<NIN, Op, kUnroll<NIN, ACC>, NT, ACC>;
    else return fold_kernel<NIN, Op, kUnroll<NIN, ACC>, NT, ACC>;
}
template <int NIN, class Op, bool NT, bool ACC>
BatchFn batch_ptr() { return batch_kernel<NIN, Op, kUnroll<NIN, ACC>, NT, ACC>; }

template <bool NT, bool FULL>
struct CopyOf {
    template <int NR>
    struct At {
        static FoldFn get() {
            if constexpr (FULL) return copy_full_kernel<NR, kCopyUnroll, NT>;
            else return copy_kernel<NR, kCopyUnroll, NT>;
        }
    };
};

// Kernel for nin = 1..16 ranks; Make<NIN>::get() names the instantiation.
template <template <int> class Make, class Fn>
Fn pick_nin(int nin) {
    switch (nin) {
        case 1: return Make<1>::get();
        case 2: return Make<2>::get();
        case 3: return Make<3>::get();
        case 4: return Make<4>::get();
        case 5: return Make<5>::get();
        case 6: return Make<6>::get();
        case 7: return Make<7>::get();
        case 8: return Make<8>::get();
        case 9: return Make<9>::get();
        case 10: return Make<10>::get();
        case 11: return Make<11>::get();
        case 12: return Make<12>::get();
        case 13: return Make<13>::get();
        case 14: return Make<14>::get();
        case 15: return Make<15>::get();
        case 16: return Make<16>::get();
        default: return nullptr;
    }
}

template <bool NT, bool FULL>
FoldFn pick_copy(int nranks) {
    return pick_nin<CopyOf<NT, FULL>::template At, FoldFn>(nranks);
}

template <class Op, bool NT, bool ACC, bool FULL, bool U1>
struct FoldOf {
    template <int NIN>
    struct At {
        static FoldFn get() { return fold_ptr<NIN, Op, NT, ACC, FULL, U1>(); }
    };
};
template <class Op, bool NT, bool ACC>
struct BatchOf {
    template <int NIN>
    struct At {
        static BatchFn get() { return batch_ptr<NIN, Op, NT, ACC>(); }
    };
};

// Accumulators exist for Sum and Mean only (validation refuses Max).
template <bool NT, bool ACC, bool FULL, bool U1>
FoldFn pick_fold_op(int dtype, int op, int nin) {
    if (dtype == RC_F32) {
        if (op == RC_MAX) {
            if constexpr (ACC) return nullptr;
            else return pick_nin<FoldOf<OpMaxF32, NT, false, FULL, U1>::template At, FoldFn>(nin);
        }
        return pick_nin<FoldOf<OpSumF32, NT, ACC, FULL, U1>::template At, FoldFn>(nin);
    }
    if (op == RC_MAX) {
        if constexpr (ACC) return nullptr;
        else return pick_nin<FoldOf<OpMaxI32, NT, false, FULL, U1>::template At, FoldFn>(nin);
    }
    return pick_nin<FoldOf<OpSumI32, NT, ACC, FULL, U1>::template At, FoldFn>(nin);
}

template <bool NT, bool ACC>
BatchFn pick_batch_op(int dtype, int op, int nin) {
    if (dtype == RC_F32) {
        if (op == RC_MAX) {
            if constexpr (ACC) return nullptr;
            else return pick_nin<BatchOf<OpMaxF32, NT, false>::template At, BatchFn>(nin);
        }
        return pick_nin<BatchOf<OpSumF32, NT, ACC>::template At, BatchFn>(nin);
    }
    if (op == RC_MAX) {
        if constexpr (ACC) return nullptr;
        else return pick_nin<BatchOf<OpMaxI32, NT, false>::template At, BatchFn>(nin);
    }
    return pick_nin<BatchOf<OpSumI32, NT, ACC>::template At, BatchFn>(nin);
}

template <bool NT>
struct CopyBatchOf {
    template <int NR>
    struct At {
        static BatchFn get() { return copy_batch_kernel<NR, kCopyUnroll, NT>; }
    };
};

using CopyArgsFn = void (*)(CopyArgs);
template <bool NT, bool FULL>
struct CopyArgsOf {
    template <int NR>
    struct At {
        static CopyArgsFn get() {
            if constexpr (FULL) return copy_args_full_kernel<NR, kCopyUnroll, NT>;
            else return copy_args_kernel<NR, kCopyUnroll, NT>;
        }
    };
};

template <bool NT, bool FULL>
FoldFn pick_fold_any(int dtype, int op, int nin, bool acc, bool u1) {
    if (acc) return pick_fold_op<NT, true, FULL, false>(dtype, op, nin);
    if constexpr (FULL) {
        if (u1) return pick_fold_op<NT, false, true, true>(dtype, op, nin);
    }
    return pick_fold_op<NT, false, FULL, false>(dtype, op, nin);
}
template <bool NT>
BatchFn pick_batch_any(int dtype, int op, int nin, bool acc) {
    return acc ? pick_batch_op<NT, true>(dtype, op, nin) : pick_batch_op<NT, false>(dtype, op, nin);
}

}  // namespace

hipError_t launch_jobs(const LaunchPlan& p, hipStream_t stream) {
    const bool nt = p.args.nontemporal != 0;
    const bool full = p.args.full_tiles != 0;
    FoldFn fn;
    if (p.args.in_mode == kInCopy) {
        const int nr = p.args.nranks;
        fn = nt ? (full ? pick_copy<true, true>(nr) : pick_copy<true, false>(nr))
                : (full ? pick_copy<false, true>(nr) : pick_copy<false, false>(nr));
    } else {
        // the one-vector whole-tile all-reduce of 4-7 ranks (see plan)
        const bool mid = !p.acc && p.nin >= 4 && p.nin < 8;
        const bool u1 = full && mid && p.unroll == 1;
        if (mid && !full && p.unroll != 2) return hipErrorInvalidValue;  // no general kernel with one vector
        fn = nt ? (full ? pick_fold_any<true, true>(p.dtype, p.op, p.nin, p.acc, u1)
                        : pick_fold_any<true, false>(p.dtype, p.op, p.nin, p.acc, false))
                : (full ? pick_fold_any<false, true>(p.dtype, p.op, p.nin, p.acc, u1)
                        : pick_fold_any<false, false>(p.dtype, p.op, p.nin, p.acc, false));
    }
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(p.grid, p.grid_y), dim3(kBlock), p.lds_bytes, stream, p.args);
    return hipGetLastError();
}

hipError_t launch_batch(const BatchJob* jobs, const int32_t* group_job, const void* const* ptrs,
                        const BatchPlan& p, hipStream_t stream) {
    const bool nt = p.nontemporal != 0;
    BatchFn fn;
    if (p.copy) fn = nt ? pick_nin<CopyBatchOf<true>::template At, BatchFn>(p.nout)
                        : pick_nin<CopyBatchOf<false>::template At, BatchFn>(p.nout);
    else fn = nt ? pick_batch_any<true>(p.dtype, p.op, p.nranks, p.acc)
                 : pick_batch_any<false>(p.dtype, p.op, p.nranks, p.acc);
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
    const bool nt = p.nontemporal != 0;
    const bool full = p.full_tiles;
    CopyArgsFn fn = nt ? (full ? pick_nin<CopyArgsOf<true, true>::template At, CopyArgsFn>(p.nout)
                               : pick_nin<CopyArgsOf<true, false>::template At, CopyArgsFn>(p.nout))
                       : (full ? pick_nin<CopyArgsOf<false, true>::template At, CopyArgsFn>(p.nout)
                               : pick_nin<CopyArgsOf<false, false>::template At, CopyArgsFn>(p.nout));
    if (!fn) return hipErrorInvalidValue;
    CopyArgs a{};
    for (size_t i = 0; i < p.ptrs.size(); ++i) a.ptrs[i] = p.ptrs[i];
    a.len = p.jobs[0].len;
    a.tile_elems = p.tile_elems;
    for (size_t j = 0; j < p.jobs.size(); ++j) {
        if (p.jobs[j].len != a.len) return hipErrorInvalidValue;  // equal lengths only
        a.phase[j] = (uint8_t)p.jobs[j].phase;
    }
    hipLaunchKernelGGL(fn, dim3(p.grid, p.grid_y), dim3(kBlock), p.lds_bytes, stream, a);
    return hipGetLastError();
}

}  // namespace rc
