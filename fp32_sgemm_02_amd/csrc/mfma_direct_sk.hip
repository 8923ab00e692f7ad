// mfma_direct_sk.hip -- stream-K launchers of the direct-load tiles (the
// persistent runs and the fixup of direct_kernel.hpp, MODE 1 and 2), one per
// entry of direct_tiles.inc and of direct_ta_tiles.inc in the same order
// (none for tiles that do not offer stream-K).  Kept apart from the tile
// tables so that the two compile in parallel.
#include "direct_kernel.hpp"

namespace sg {

const LaunchFn *mfma_direct_sk_launchers(int *count) {
    static const LaunchFn fns[] = {
#define DIRECT_TILE(BM, BN, BK, WM, WN, NBUF, EDGES, KG, EFF) \
    streamk_launcher<BM, BN, BK, WM, WN, NBUF, EDGES, KG, false>(),
#include "direct_tiles.inc"
#undef DIRECT_TILE
    };
    *count = sizeof(fns) / sizeof(fns[0]);
    return fns;
}

const LaunchFn *mfma_direct_ta_sk_launchers(int *count) {
    static const LaunchFn fns[] = {
#define DIRECT_TILE(BM, BN, BK, WM, WN, NBUF, EDGES, KG, EFF) \
    streamk_launcher<BM, BN, BK, WM, WN, NBUF, EDGES, KG, true>(),
#include "direct_ta_tiles.inc"
#undef DIRECT_TILE
    };
    *count = sizeof(fns) / sizeof(fns[0]);
    return fns;
}

}  // namespace sg
