// Reduction and fan-out kernels for gfx950 (CDNA4, wave64): device code shared
// by the kernel translation units, each of which instantiates one family.
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
// elements split into a scalar head (until its reference stream is 16-byte
// aligned), a body of 16-byte vectors, and a scalar tail (fewer than 4
// elements); head and tail are done by the lanes of the job's first tile
// (tiling.h).  Streams that are not aligned like the reference are accessed
// with the same 16-byte instructions at 4-byte aligned addresses, which the
// HSA runtime's unaligned access mode serves.  Each element is read and
// written by exactly one lane, and there are no atomics, so the summation
// order is the documented one whatever the grid.
#pragma once

#include <hip/hip_runtime.h>

#include "rc_internal.h"

namespace rc {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// the memory view of a 16-byte vector: 4-byte alignment, so that streams off
// the reference's 16-byte grid use the same instructions
typedef uint32_t u32x4m __attribute__((ext_vector_type(4), aligned(4)));

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

// ---------------------------------------------------------------- operators
// Each operator works on raw 32-bit patterns.

struct OpSumF32 {
    static constexpr bool kCanMean = true;
    __device__ __forceinline__ static uint32_t apply(uint32_t a, uint32_t b) { return as_u(as_f(a) + as_f(b)); }
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
        const int32_t x = (int32_t)a, y = (int32_t)b;
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
        const float x = as_f(a), y = as_f(b);
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
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4m*>(p));
    else return *reinterpret_cast<const u32x4m*>(p);
}
template <bool NT>
__device__ __forceinline__ void st4(uint32_t* p, u32x4 v) {
    const u32x4m w = v;
    if constexpr (NT) __builtin_nontemporal_store(w, reinterpret_cast<u32x4m*>(p));
    else *reinterpret_cast<u32x4m*>(p) = w;
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

// One scalar element.  With ACC, operand k is acc[k] + in[k] (an accumulator
// plus the last gradient, one add per element with the reduction's Sum),
// added before the fold.
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

// Tile lt of a job of `len` elements: its vectors in rounds of U per lane,
// and on tile 0 the job's scalar head and tail.
template <int NIN, int NR, class Op, int U, bool NT, bool ACC, class OutF>
__device__ __forceinline__ void job_tile(const uint32_t* const (&in)[NIN], const uint32_t* const (&ac)[NIN],
                                         const OutF& out, uint32_t mask, int64_t len, uint8_t phase, int64_t lt,
                                         int64_t te, bool mean) {
    const JobSplit s = job_split(len, phase, te);
    int64_t v0, v1;
    tile_vectors(s, lt, &v0, &v1);
    constexpr int64_t kStep = (int64_t)kBlock * U;
    for (int64_t vb = v0; vb < v1; vb += kStep) {
        const int64_t off = s.head + vb * kVec;
        if (v1 - vb >= kStep) vec_round<NIN, NR, Op, U, NT, ACC, true>(in, ac, off, 0, out, mask, mean);
        else vec_round<NIN, NR, Op, U, NT, ACC, false>(in, ac, off, (uint32_t)(v1 - vb), out, mask, mean);
    }
    if (lt == 0) {
        const int64_t lane = threadIdx.x;
        if (lane < scalars_of(s, len)) element<NIN, NR, Op, NT, ACC>(in, ac, scalar_elem(s, lane), out, mask, mean);
    }
}

// ---------------------------------------------------------------- kernels

// Tile lt of fold job c: operand k is rank fold_rank(c, k) at element
// c*in_stride (with ACC, plus that rank's accumulator at the same element).
template <int NIN, class Op, int U, bool NT, bool ACC>
__device__ __forceinline__ void fold_tile(const JobArgs& a, int c, int lt) {
    const int64_t len = job_len(a.n, a.seg, c);
    const int64_t ioff = (int64_t)c * a.in_stride;
    const uint32_t* in[NIN];
    const uint32_t* ac[NIN];
#pragma unroll
    for (int k = 0; k < NIN; ++k) {
        const int r = fold_rank(c, k, NIN);
        in[k] = static_cast<const uint32_t*>(a.in[r]) + ioff;
        ac[k] = ACC ? static_cast<const uint32_t*>(a.acc[r]) + ioff : nullptr;
    }
    const Outs<NIN> out = outs_of<NIN>(a.out, (int64_t)c * a.out_stride);
    job_tile<NIN, NIN, Op, U, NT, ACC>(in, ac, out, out_mask_of(a.out_mode, a.out_mask, c), len, a.phase[c], lt,
                                       a.tile_elems, a.mean != 0);
}

// Tile lt of copy job c: in[c] at element c*in_stride, copied bit for bit to
// the outputs of up to NR ranks.
template <int NR, int U, bool NT>
__device__ __forceinline__ void copy_tile(const JobArgs& a, int c, int lt) {
    const int64_t len = job_len(a.n, a.seg, c);
    const uint32_t* in[1] = {static_cast<const uint32_t*>(a.in[c]) + (int64_t)c * a.in_stride};
    const uint32_t* none[1] = {nullptr};
    const Outs<NR> out = outs_of<NR>(a.out, (int64_t)c * a.out_stride);
    job_tile<1, NR, OpSumI32, U, NT, false>(in, none, out, out_mask_of(a.out_mode, a.out_mask, c), len, a.phase[c],
                                            lt, a.tile_elems, false);
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
        const int r = fold_rank(c, k, NIN);
        in[k] = static_cast<const uint32_t*>(a.in[r]) + ioff;
        ac[k] = ACC ? static_cast<const uint32_t*>(a.acc[r]) + ioff : nullptr;
    }
    const Outs<NIN> out = outs_of<NIN>(a.out, (int64_t)c * a.out_stride + e0);
    vec_round<NIN, NIN, Op, U, NT, ACC, true>(in, ac, 0, 0, out, out_mask_of(a.out_mode, a.out_mask, c),
                                             a.mean != 0);
}

// A split fold's edge tile: workgroup x < a.edges of job c does the job's
// tile skipped_tile(x, 1, a.interior) (its tile 0, with the scalars, or one
// past its interior) on the general path, from the job's first element.
template <int NIN, class Op, int U, bool NT>
__device__ __forceinline__ void table_edge_tile(const FoldTable& a, int c, int x) {
    constexpr int T = kBlock * kVec * U;
    const int64_t lt = skipped_tile(x, 1, a.interior);
    if (lt >= tiles_of(a.len[c], a.phase[c], T)) return;
    const uint32_t* in[NIN];
    const uint32_t* none[NIN];
#pragma unroll
    for (int k = 0; k < NIN; ++k) {
        in[k] = static_cast<const uint32_t*>(a.in[c][k]) - a.out_off[c];
        none[k] = nullptr;
    }
    const Outs<NIN> out = outs_of<NIN>(a.out, (int64_t)c * a.out_stride);
    job_tile<NIN, NIN, Op, U, NT, false>(in, none, out, a.mask[c], a.len[c], a.phase[c], lt, T, a.mean != 0);
}

// The whole-tile fold over a FoldTable: workgroup (x, y) = (tile, job); job
// c's inputs start at in[c][k] and its outputs at its place.  EDGES (a split
// fold): the first a.edges workgroups of each job do its edge tiles
// (table_edge_tile), dispatched first so that their latency overlaps the
// interior's, and the rest the interior, whose outputs start out_off[c]
// elements into the job.  ACC: operand k is in[c][kAccSlot + k] (its
// accumulator) plus in[c][k].
template <int NIN, class Op, int U, bool NT, bool EDGES, bool ACC = false>
__device__ __forceinline__ void table_round(const FoldTable& a) {
    static_assert(!ACC || (NIN <= kAccSlot && !EDGES), "accumulators: up to kAccSlot ranks, whole tiles");
    const int c = blockIdx.y;
    int64_t x = blockIdx.x;
    if constexpr (EDGES) {
        if (x < a.edges) {
            table_edge_tile<NIN, Op, U, NT>(a, c, (int)x);
            return;
        }
        x -= a.edges;
    }
    const int64_t e0 = x * (kBlock * kVec * U);
    const uint32_t* in[NIN];
    const uint32_t* ac[NIN];
#pragma unroll
    for (int k = 0; k < NIN; ++k) {
        in[k] = static_cast<const uint32_t*>(a.in[c][k]) + e0;
        ac[k] = ACC ? static_cast<const uint32_t*>(a.in[c][kAccSlot + k]) + e0 : nullptr;
    }
    // only a split fold's interior starts off the job's first element
    const int64_t ooff = EDGES ? a.out_off[c] : 0;
    const Outs<NIN> out = outs_of<NIN>(a.out, (int64_t)c * a.out_stride + ooff + e0);
    vec_round<NIN, NIN, Op, U, NT, ACC, true>(in, ac, 0, 0, out, a.mask[c], a.mean != 0);
}

template <int NIN, class Op, int U, bool NT>
__global__ __launch_bounds__(kBlock) void fold_table_kernel(FoldTable a) {
    table_round<NIN, Op, U, NT, false>(a);
}

// Whole-tile folds with accumulators of up to kAccSlot ranks (a gradient
// sync that adds the last microbatch's gradients into the accumulators).
template <int NIN, class Op, int U, bool NT>
__global__ __launch_bounds__(kBlock) void fold_table_acc_kernel(FoldTable a) {
    table_round<NIN, Op, U, NT, false, true>(a);
}

// The edge form: a split fold (the first a.edges workgroups of each job do
// its edge tiles).
template <int NIN, class Op, int U, bool NT>
__global__ __launch_bounds__(kBlock) void fold_table_edges_kernel(FoldTable a) {
    table_round<NIN, Op, U, NT, true>(a);
}

// One whole-tile round of a launch in which some written output starts its
// job off a 64-byte write burst (tiling.h): in[k] and out(o) are at the
// tile's first element.  Outputs on a burst boundary are written from
// registers as by vec_round; the others over burst-aligned ranges, from the
// round's values staged in LDS (at least shift_lds_bytes(U): the dynamic
// allocation that caps occupancy) behind the pre_vectors folded ahead of the
// tile.  A tile writes up to kBurstElems - 1 elements before its own, which
// the previous tile reads as inputs if an output aliases an input: the
// planners never pick this path for calls in place.  NIN = 1 with OpSumI32
// is a copy.
template <int NIN, int NR, class Op, int U, bool NT>
__device__ __forceinline__ void shifted_round(const uint32_t* const (&in)[NIN], const Outs<NR>& out,
                                              uint32_t mask, bool first, bool last, bool mean) {
    extern __shared__ uint32_t stage[];
    constexpr int T = kBlock * kVec * U;
    const int lane = (int)threadIdx.x;
    int mmax = 0;
#pragma unroll
    for (int o = 0; o < NR; ++o)
        if ((mask >> o) & 1u) mmax = max(mmax, burst_offset(reinterpret_cast<uintptr_t>(out(o))));
    const int npre = pre_vectors(mmax, first);
    u32x4 x[U][NIN];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < NIN; ++k) x[u][k] = ld4<NT>(in[k] + (size_t)((u * kBlock + lane) * kVec));
    const bool pre = lane < npre;
    u32x4 xp[NIN];
    if (pre) {
#pragma unroll
        for (int k = 0; k < NIN; ++k) xp[k] = ld4<NT>(in[k] - (int64_t)(npre - lane) * kVec);
    }
    out.pin();
    u32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        acc[u] = fold<NIN, Op>(x[u]);
        if constexpr (Op::kCanMean) {
            if (mean) acc[u] = mean4<NIN>(acc[u]);
        }
    }
    uint32_t shifted = 0;
#pragma unroll
    for (int o = 0; o < NR; ++o) {
        if (!((mask >> o) & 1u)) continue;
        uint32_t* p = out(o);
        if (burst_offset(reinterpret_cast<uintptr_t>(p))) {
            shifted |= 1u << o;
            continue;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) st4<NT>(p + (size_t)((u * kBlock + lane) * kVec), acc[u]);
    }
    if (!shifted) return;
    // stage[j]: the value of element e0 - kBurstElems + j (e0: the tile's first)
#pragma unroll
    for (int u = 0; u < U; ++u)
        *reinterpret_cast<u32x4*>(&stage[kBurstElems + (u * kBlock + lane) * kVec]) = acc[u];
    if (pre) {
        u32x4 ap = fold<NIN, Op>(xp);
        if constexpr (Op::kCanMean) {
            if (mean) ap = mean4<NIN>(ap);
        }
        *reinterpret_cast<u32x4*>(&stage[kBurstElems - (npre - lane) * kVec]) = ap;
    }
    __syncthreads();
#pragma unroll
    for (int o = 0; o < NR; ++o) {
        if (!((shifted >> o) & 1u)) continue;
        uint32_t* p = out(o);
        const int m = burst_offset(reinterpret_cast<uintptr_t>(p));
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int w = (u * kBlock + lane) * kVec;  // the vector's first element in [e0 - m, e0 - m + T)
            const u32x4 v = *reinterpret_cast<const u32x4m*>(&stage[kBurstElems - m + w]);
            const int lo = shifted_first(first, w, m);
            if (lo == 0) {
                st4<NT>(p + (int64_t)(w - m), v);
            } else {
#pragma unroll
                for (int i = 0; i < kVec; ++i)
                    if (i >= lo) st1<NT>(p + (int64_t)(w - m + i), v[i]);
            }
        }
        if (shifted_tail(last, m, lane)) st1<NT>(p + (T - m + lane), stage[kBurstElems + T - m + lane]);
    }
}

// The whole-tile fold over a FoldTable with outputs shifted onto their
// 64-byte bursts (shifted_round); tiles go to the XCDs in groups of
// consecutive ones (xcd_group_tile).
template <int NIN, class Op, int U, bool NT, bool EDGES>
__device__ __forceinline__ void table_shift_round(const FoldTable& a) {
    constexpr int T = kBlock * kVec * U;
    const int c = blockIdx.y;
    int64_t x = blockIdx.x;
    int64_t nx = gridDim.x;
    if constexpr (EDGES) {
        if (x < a.edges) {
            table_edge_tile<NIN, Op, U, NT>(a, c, (int)x);
            return;
        }
        x -= a.edges;
        nx = a.interior;
    }
    const int64_t xt = xcd_group_tile(x, nx);
    const int64_t e0 = xt * T;
    const uint32_t* in[NIN];
#pragma unroll
    for (int k = 0; k < NIN; ++k) in[k] = static_cast<const uint32_t*>(a.in[c][k]) + e0;
    const int64_t ooff = EDGES ? a.out_off[c] : 0;
    const Outs<NIN> out = outs_of<NIN>(a.out, (int64_t)c * a.out_stride + ooff + e0);
    shifted_round<NIN, NIN, Op, U, NT>(in, out, a.mask[c], xt == 0, xt == nx - 1, a.mean != 0);
}

template <int NIN, class Op, int U, bool NT>
__global__ __launch_bounds__(kBlock) void fold_table_shift_kernel(FoldTable a) {
    table_shift_round<NIN, Op, U, NT, false>(a);
}

template <int NIN, class Op, int U, bool NT>
__global__ __launch_bounds__(kBlock) void fold_table_shift_edges_kernel(FoldTable a) {
    table_shift_round<NIN, Op, U, NT, true>(a);
}

template <int NR, int U, bool NT>
__global__ __launch_bounds__(kBlock) void copy_full_kernel(JobArgs a) {
    const int c = blockIdx.y;
    const int64_t e0 = (int64_t)blockIdx.x * (kBlock * kVec * U);
    const uint32_t* in[1] = {static_cast<const uint32_t*>(a.in[c]) + (int64_t)c * a.in_stride + e0};
    const uint32_t* none[1] = {nullptr};
    const Outs<NR> out = outs_of<NR>(a.out, (int64_t)c * a.out_stride + e0);
    vec_round<1, NR, OpSumI32, U, NT, false, true>(in, none, 0, 0, out, out_mask_of(a.out_mode, a.out_mask, c),
                                                   false);
}

// copy_full_kernel with outputs shifted onto their 64-byte bursts
// (shifted_round, tiles grouped per XCD).
template <int NR, int U, bool NT>
__global__ __launch_bounds__(kBlock) void copy_full_shift_kernel(JobArgs a) {
    constexpr int T = kBlock * kVec * U;
    const int c = blockIdx.y;
    const int64_t xt = xcd_group_tile(blockIdx.x, gridDim.x);
    const int64_t e0 = xt * T;
    const uint32_t* in[1] = {static_cast<const uint32_t*>(a.in[c]) + (int64_t)c * a.in_stride + e0};
    const Outs<NR> out = outs_of<NR>(a.out, (int64_t)c * a.out_stride + e0);
    shifted_round<1, NR, OpSumI32, U, NT>(in, out, out_mask_of(a.out_mode, a.out_mask, c), xt == 0,
                                          xt == (int64_t)gridDim.x - 1, false);
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
        const int c = job_of(a.tile_prefix, t);
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
        const int c = job_of(a.tile_prefix, t);
        copy_tile<NR, U, NT>(a, c, t - a.tile_prefix[c]);
    }
}

// Batched all-reduce over a job table in device memory (find_job, tiling.h).
template <int NIN, class Op, int U, bool NT, bool ACC>
__global__ __launch_bounds__(kBlock) void batch_kernel(BatchArgs a) {
    constexpr int kPtrs = (ACC ? 3 : 2) * NIN;
    constexpr int kOut = (ACC ? 2 : 1) * NIN;
    for (int64_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
        const int j = find_job(a.jobs, a.group_job, a.ngroups, a.njobs, t);
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
        job_tile<NIN, NIN, Op, U, NT, ACC>(in, ac, out, (1u << NIN) - 1u, jb.len, (uint8_t)jb.phase,
                                           t - jb.tile_begin, a.tile_elems, a.mean != 0);
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
    job_tile<1, NR, OpSumI32, U, NT, false>(in, none, out, (1u << NR) - 1u, jb.len, (uint8_t)jb.phase, lt,
                                            a.tile_elems, false);
}

template <int NR, int U, bool NT>
__global__ __launch_bounds__(kBlock) void copy_batch_kernel(BatchArgs a) {
    if (a.grid_2d) {
        const int j = blockIdx.y;
        const BatchJob jb = a.jobs[j];
        if (blockIdx.x < tiles_of(jb.len, (uint8_t)jb.phase, a.tile_elems)) copy_job_tile<NR, U, NT>(a, j, blockIdx.x);
        return;
    }
    for (int64_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
        const int j = find_job(a.jobs, a.group_job, a.ngroups, a.njobs, t);
        copy_job_tile<NR, U, NT>(a, j, t - a.jobs[j].tile_begin);
    }
}

// A copy batch whose table travels in the kernel arguments: job j =
// blockIdx.y copies ptrs[j*(1+NR)] to the next NR pointers; every job has
// len elements.
template <int NR, int U, bool NT>
__global__ __launch_bounds__(kBlock) void copy_args_kernel(CopyArgs a) {
    const int j = blockIdx.y;
    const uint8_t phase = a.phase[j];
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

// copy_args_full_kernel with outputs shifted onto their 64-byte bursts.
template <int NR, int U, bool NT>
__global__ __launch_bounds__(kBlock) void copy_args_full_shift_kernel(CopyArgs a) {
    constexpr int T = kBlock * kVec * U;
    const void* const* tp = a.ptrs + blockIdx.y * (1 + NR);
    const int64_t xt = xcd_group_tile(blockIdx.x, gridDim.x);
    const int64_t e0 = xt * T;
    const uint32_t* in[1] = {static_cast<const uint32_t*>(tp[0]) + e0};
    const Outs<NR> out = outs_of<NR>(const_cast<void* const*>(tp + 1), e0);
    shifted_round<1, NR, OpSumI32, U, NT>(in, out, 0xFFFFFFFFu >> (32 - NR), xt == 0,
                                          xt == (int64_t)gridDim.x - 1, false);
}

// ---------------------------------------------------------------- dispatch helpers

// Vectors per lane per round: about eight 16-byte loads in flight per lane,
// counting an accumulator's loads with the operands'.
template <int NIN, bool ACC>
constexpr int kUnroll = unroll_for(ACC ? 2 * NIN : NIN);

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

}  // namespace
}  // namespace rc
