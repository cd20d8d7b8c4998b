// block_scan_k.hip -- the block-affine and cumulative-product kernels for one
// block size k other than 8, chosen at compile time with -DMGS_ROWS_K=<k>
// (the build compiles this file once for each of k = 1, 2, 4, 16, in
// parallel).  The device code is in block_core.hpp; the entry points that
// dispatch to it are in block_scan.hip.
#include <hip/hip_runtime.h>

#include "block_core.hpp"

#ifndef MGS_ROWS_K
#error "compile with -DMGS_ROWS_K=<k>, k in {1, 2, 4, 16}"
#endif
static_assert(MGS_ROWS_K == 1 || MGS_ROWS_K == 2 || MGS_ROWS_K == 4 || MGS_ROWS_K == 16,
              "block_scan_k.hip serves k = 1, 2, 4, 16 (k = 8 is in block_scan.hip)");

namespace mgs {

template <>
void launch_blk<MGS_ROWS_K>(BlkOp op, const BlockGeom &g, const BlkArgs &a, hipStream_t s)
{
    launch_blk_impl<MGS_ROWS_K>(op, g, a, s);
}

}  // namespace mgs
