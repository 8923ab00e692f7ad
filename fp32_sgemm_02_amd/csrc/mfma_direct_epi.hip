// mfma_direct_epi.hip -- fused-epilogue launchers of the direct-load
// tiles for untransposed A (bias and activation applied in the kernel's own
// epilogue), one per entry of direct_tiles.inc, in the same order.  Kept
// apart from the tile table so that the two compile in parallel.
#include "direct_kernel.hpp"

namespace sg {

const LaunchFn *mfma_direct_epi_launchers(int *count) {
    static const LaunchFn fns[] = {
#define DIRECT_TILE(BM, BN, BK, WM, WN, NBUF, EDGES, KG, EFF) \
    &launch_direct_epi<BM, BN, BK, WM, WN, NBUF, KG, false, EDGES>,
#include "direct_tiles.inc"
#undef DIRECT_TILE
    };
    *count = sizeof(fns) / sizeof(fns[0]);
    return fns;
}

}  // namespace sg
