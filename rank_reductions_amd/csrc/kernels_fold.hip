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

// General folds (JobArgs), and whole-tile folds with accumulators of more
// than kAccSlot ranks; unroll kUnroll.
template <class Op, bool ACC, bool FULL>
struct FoldOf {
    template <int NIN>
    struct At {
        static FoldFn get() {
            if constexpr (FULL && NIN <= kAccSlot) return nullptr;  // fold_table_acc_kernel
            else if constexpr (FULL) return fold_full_kernel<NIN, Op, kUnroll<NIN, ACC>, kNt, ACC>;
            else return fold_kernel<NIN, Op, kUnroll<NIN, ACC>, kNt, ACC>;
        }
    };
};

template <bool FULL>
FoldFn pick(int op, bool acc, int nin) {
    if constexpr (FULL) {
        // whole-tile folds without accumulators run fold_table_kernel, and
        // those with accumulators of up to kAccSlot ranks fold_table_acc_kernel
        if (!acc || op == RC_MAX) return nullptr;
        return pick_nin<FoldOf<SumOp, true, true>::template At, FoldFn>(nin);
    } else {
        if (op == RC_MAX) return acc ? nullptr : pick_nin<FoldOf<MaxOp, false, false>::template At, FoldFn>(nin);
        if (acc) return pick_nin<FoldOf<SumOp, true, false>::template At, FoldFn>(nin);
        return pick_nin<FoldOf<SumOp, false, false>::template At, FoldFn>(nin);
    }
}

// U1: the whole-tile all-reduce of 4-7 ranks with one vector per lane (the
// planner halves its tiles); every other whole-tile fold uses kUnroll.
// SHIFT: the kernel for launches with outputs off a 64-byte write burst;
// EDGES: the form of split folds (kUnroll only).
template <class Op, bool U1, bool SHIFT, bool EDGES>
struct TableOf {
    template <int NIN>
    struct At {
        static constexpr int kU = (U1 && NIN >= 4 && NIN < 8) ? 1 : kUnroll<NIN, false>;
        static FoldTableFn get() {
            if constexpr (SHIFT && EDGES) return fold_table_shift_edges_kernel<NIN, Op, kU, kNt>;
            else if constexpr (SHIFT) return fold_table_shift_kernel<NIN, Op, kU, kNt>;
            else if constexpr (EDGES) return fold_table_edges_kernel<NIN, Op, kU, kNt>;
            else return fold_table_kernel<NIN, Op, kU, kNt>;
        }
    };
};

template <class Op, bool SHIFT>
FoldTableFn pick_table_op(bool u1, bool edges, int nin) {
    if (edges) return u1 ? nullptr : pick_nin<TableOf<Op, false, SHIFT, true>::template At, FoldTableFn>(nin);
    return u1 ? pick_nin<TableOf<Op, true, SHIFT, false>::template At, FoldTableFn>(nin)
              : pick_nin<TableOf<Op, false, SHIFT, false>::template At, FoldTableFn>(nin);
}

FoldTableFn pick_table(int op, bool u1, bool shift, bool edges, int nin) {
    if (op == RC_MAX)
        return shift ? pick_table_op<MaxOp, true>(u1, edges, nin) : pick_table_op<MaxOp, false>(u1, edges, nin);
    return shift ? pick_table_op<SumOp, true>(u1, edges, nin) : pick_table_op<SumOp, false>(u1, edges, nin);
}

// Whole-tile folds with accumulators of up to kAccSlot ranks (Sum; Mean is
// Sum with the table's mean flag).
template <int NIN>
struct AccTableAt {
    static FoldTableFn get() {
        if constexpr (NIN <= kAccSlot) return fold_table_acc_kernel<NIN, SumOp, kUnroll<NIN, true>, kNt>;
        else return nullptr;
    }
};

FoldTableFn pick_acc_table(int op, int nin) {
    return op == RC_MAX ? nullptr : pick_nin<AccTableAt, FoldTableFn>(nin);
}

FoldFn pick_any(int op, bool acc, bool full, bool u1, int nin) {
    (void)u1;
    return full ? pick<true>(op, acc, nin) : pick<false>(op, acc, nin);
}

}  // namespace

#if RC_KDT == RC_F32 && RC_KNT
FoldFn fold_fn_f32_nt(int op, bool acc, bool full, bool u1, int nin) { return pick_any(op, acc, full, u1, nin); }
FoldTableFn fold_table_fn_f32_nt(int op, bool u1, bool shift, bool edges, int nin) {
    return pick_table(op, u1, shift, edges, nin);
}
FoldTableFn fold_table_acc_fn_f32_nt(int op, int nin) { return pick_acc_table(op, nin); }
#elif RC_KDT == RC_F32
FoldFn fold_fn_f32_cached(int op, bool acc, bool full, bool u1, int nin) { return pick_any(op, acc, full, u1, nin); }
FoldTableFn fold_table_fn_f32_cached(int op, bool u1, bool shift, bool edges, int nin) {
    return pick_table(op, u1, shift, edges, nin);
}
FoldTableFn fold_table_acc_fn_f32_cached(int op, int nin) { return pick_acc_table(op, nin); }
#elif RC_KNT
FoldFn fold_fn_i32_nt(int op, bool acc, bool full, bool u1, int nin) { return pick_any(op, acc, full, u1, nin); }
FoldTableFn fold_table_fn_i32_nt(int op, bool u1, bool shift, bool edges, int nin) {
    return pick_table(op, u1, shift, edges, nin);
}
FoldTableFn fold_table_acc_fn_i32_nt(int op, int nin) { return pick_acc_table(op, nin); }
#else
FoldFn fold_fn_i32_cached(int op, bool acc, bool full, bool u1, int nin) { return pick_any(op, acc, full, u1, nin); }
FoldTableFn fold_table_fn_i32_cached(int op, bool u1, bool shift, bool edges, int nin) {
    return pick_table(op, u1, shift, edges, nin);
}
FoldTableFn fold_table_acc_fn_i32_cached(int op, int nin) { return pick_acc_table(op, nin); }
#endif

}  // namespace rc
