// Batched all-reduce kernels (the small tensors of a whole-gradient
// all-reduce or gradient sync, over a job table in device memory) for one
// cache hint, chosen at build time (RC_KNT: 1 non-temporal, 0 cached).
#include "kernels_impl.h"

#if !defined(RC_KNT)
#error "build with -DRC_KNT=<0|1>"
#endif

namespace rc {
namespace {

constexpr bool kNt = RC_KNT != 0;

template <class Op, bool ACC>
struct BatchOf {
    template <int NIN>
    struct At {
        static BatchFn get() { return batch_kernel<NIN, Op, kUnroll<NIN, ACC>, kNt, ACC>; }
    };
};

// Accumulators exist for Sum and Mean only (validation refuses Max).
template <class SumOp, class MaxOp>
BatchFn pick(int op, bool acc, int nin) {
    if (op == RC_MAX) return acc ? nullptr : pick_nin<BatchOf<MaxOp, false>::template At, BatchFn>(nin);
    if (acc) return pick_nin<BatchOf<SumOp, true>::template At, BatchFn>(nin);
    return pick_nin<BatchOf<SumOp, false>::template At, BatchFn>(nin);
}

BatchFn pick_any(int dtype, int op, bool acc, int nin) {
    return dtype == RC_F32 ? pick<OpSumF32, OpMaxF32>(op, acc, nin) : pick<OpSumI32, OpMaxI32>(op, acc, nin);
}

}  // namespace

#if RC_KNT
BatchFn batch_fn_nt(int dtype, int op, bool acc, int nin) { return pick_any(dtype, op, acc, nin); }
#else
BatchFn batch_fn_cached(int dtype, int op, bool acc, int nin) { return pick_any(dtype, op, acc, nin); }
#endif

}  // namespace rc
