// Copy kernels (broadcast, all_gather, the ring's all-gather phase,
// send/recv, all_to_all_single, the list form of all_gather) and the table
// writer of the allocation-free batched all-reduce.
#include "kernels_impl.h"

namespace rc {
namespace {

// SHIFT: the whole-tile kernel for launches with outputs off a 64-byte
// write burst.
template <bool NT, bool FULL, bool SHIFT = false>
struct CopyOf {
    template <int NR>
    struct At {
        static FoldFn get() {
            if constexpr (SHIFT) return copy_full_shift_kernel<NR, kCopyUnroll, NT>;
            else if constexpr (FULL) return copy_full_kernel<NR, kCopyUnroll, NT>;
            else return copy_kernel<NR, kCopyUnroll, NT>;
        }
    };
};

template <bool NT>
struct CopyBatchOf {
    template <int NR>
    struct At {
        static BatchFn get() { return copy_batch_kernel<NR, kCopyUnroll, NT>; }
    };
};

template <bool NT, bool FULL, bool SHIFT = false>
struct CopyArgsOf {
    template <int NR>
    struct At {
        static CopyArgsFn get() {
            if constexpr (SHIFT) return copy_args_full_shift_kernel<NR, kCopyUnroll, NT>;
            else if constexpr (FULL) return copy_args_full_kernel<NR, kCopyUnroll, NT>;
            else return copy_args_kernel<NR, kCopyUnroll, NT>;
        }
    };
};

// Writes one piece of a descriptor table (c.nwords 32-bit words) to c.dst.
__global__ __launch_bounds__(kBlock) void table_write_kernel(TableChunk c) {
    for (uint32_t i = threadIdx.x; i < c.nwords; i += kBlock) c.dst[i] = c.words[i];
}

}  // namespace

FoldFn copy_fn(bool nt, bool full, bool shift, int nr) {
    if (shift) {
        if (!full) return nullptr;
        return nt ? pick_nin<CopyOf<true, true, true>::template At, FoldFn>(nr)
                  : pick_nin<CopyOf<false, true, true>::template At, FoldFn>(nr);
    }
    if (nt) return full ? pick_nin<CopyOf<true, true>::template At, FoldFn>(nr)
                        : pick_nin<CopyOf<true, false>::template At, FoldFn>(nr);
    return full ? pick_nin<CopyOf<false, true>::template At, FoldFn>(nr)
                : pick_nin<CopyOf<false, false>::template At, FoldFn>(nr);
}

BatchFn copy_batch_fn(bool nt, int nr) {
    return nt ? pick_nin<CopyBatchOf<true>::template At, BatchFn>(nr)
              : pick_nin<CopyBatchOf<false>::template At, BatchFn>(nr);
}

CopyArgsFn copy_args_fn(bool nt, bool full, bool shift, int nr) {
    if (shift) {
        if (!full) return nullptr;
        return nt ? pick_nin<CopyArgsOf<true, true, true>::template At, CopyArgsFn>(nr)
                  : pick_nin<CopyArgsOf<false, true, true>::template At, CopyArgsFn>(nr);
    }
    if (nt) return full ? pick_nin<CopyArgsOf<true, true>::template At, CopyArgsFn>(nr)
                        : pick_nin<CopyArgsOf<true, false>::template At, CopyArgsFn>(nr);
    return full ? pick_nin<CopyArgsOf<false, true>::template At, CopyArgsFn>(nr)
                : pick_nin<CopyArgsOf<false, false>::template At, CopyArgsFn>(nr);
}

TableFn table_write_fn() { return table_write_kernel; }

}  // namespace rc
