// mfma_direct_ta.hip -- the direct-load MFMA tiles for A stored transposed
// (K x M): the tile table of the kernel templates in direct_kernel.hpp with
// A's K-slice staged k-major, for B untransposed or transposed.  Every tile
// is compiled with edges; wave tiles are 64 rows high (whole 64-row groups).
#include "direct_kernel.hpp"

namespace sg {

const TileEntry *mfma_direct_ta_tiles(int *count) {
    static const TileEntry tiles[] = {
#define DIRECT_TILE(BM, BN, BK, WM, WN, NBUF, EDGES, KG, EFF) \
    direct_entry<BM, BN, BK, WM, WN, NBUF, EDGES, KG, true>(EFF),
#include "direct_ta_tiles.inc"
#undef DIRECT_TILE
    };
    *count = sizeof(tiles) / sizeof(tiles[0]);
    return tiles;
}

}  // namespace sg
