// Fold kernels (all_reduce, reduce, reduce_scatter, the ring's first phase,
// gradient syncs with accumulators) for one element type and one cache hint,
// chosen at build time (RC_KDT: RC_F32 or RC_I32; RC_KNT: 1 non-temporal, 0
// cached), so the instantiations compile in parallel.
#include <type_traits>

#include "kernels_impl.h"

#if !defined(RC_KDT) || !defined(RC_KNT)
#error "build with -DRC_KDT=<RC_F32|RC_I32 value> -DRC_KNT=<0|1>"
#endif

namespace rc {
namespace {

constexpr bool kNt = RC_KNT != 0;
using SumOp = std::conditional_t<RC_KDT == RC_F32, OpSumF32, OpSumI32>;
using MaxOp = std::conditional_t<RC_KDT == RC_F32, OpMaxF32, OpMaxI32>;

// U1: the whole-tile all-reduce of 4-7 ranks with one vector per lane (the
// planner halves its tiles); every other launch uses kUnroll.
template <class Op, bool ACC, bool FULL, bool U1>
struct FoldOf {
    template <int NIN>
    struct At {
        static FoldFn get() {
            if constexpr (FULL && U1 && NIN >= 4 && NIN < 8 && !ACC) return fold_full_kernel<NIN, Op, 1, kNt, ACC>;
            else if constexpr (FULL) return fold_full_kernel<NIN, Op, kUnroll<NIN, ACC>, kNt, ACC>;
            else return fold_kernel<NIN, Op, kUnroll<NIN, ACC>, kNt, ACC>;
        }
    };
};

template <bool FULL, bool U1>
FoldFn pick(int op, bool acc, int nin) {
    if (op == RC_MAX) return acc ? nullptr : pick_nin<FoldOf<MaxOp, false, FULL, U1>::template At, FoldFn>(nin);
    if (acc) return pick_nin<FoldOf<SumOp, true, FULL, false>::template At, FoldFn>(nin);
    return pick_nin<FoldOf<SumOp, false, FULL, U1>::template At, FoldFn>(nin);
}

FoldFn pick_any(int op, bool acc, bool full, bool u1, int nin) {
    if (!full) return pick<false, false>(op, acc, nin);
    if (u1 && !acc) return pick<true, true>(op, acc, nin);
    return pick<true, false>(op, acc, nin);
}

}  // namespace

#if RC_KDT == RC_F32 && RC_KNT
FoldFn fold_fn_f32_nt(int op, bool acc, bool full, bool u1, int nin) { return pick_any(op, acc, full, u1, nin); }
#elif RC_KDT == RC_F32
FoldFn fold_fn_f32_cached(int op, bool acc, bool full, bool u1, int nin) { return pick_any(op, acc, full, u1, nin); }
#elif RC_KNT
FoldFn fold_fn_i32_nt(int op, bool acc, bool full, bool u1, int nin) { return pick_any(op, acc, full, u1, nin); }
#else
FoldFn fold_fn_i32_cached(int op, bool acc, bool full, bool u1, int nin) { return pick_any(op, acc, full, u1, nin); }
#endif

}  // namespace rc
