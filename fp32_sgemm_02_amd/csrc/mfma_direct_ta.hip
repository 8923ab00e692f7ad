// mfma_direct_ta.hip -- the direct-load MFMA tiles for A stored transposed
// (K x M): the tile table of the kernel templates in direct_kernel.hpp with
// A's K-slice staged k-major, for B untransposed or transposed.  Every tile
// is compiled with edges; wave tiles are 64 rows high (whole 64-row groups).
#include "direct_kernel.hpp"

namespace sg {

const TileEntry *mfma_direct_ta_tiles(int *count) {
    static const TileEntry tiles[] = {
        // argument: % of the fp32 peak expected at 4096^3 (the untransposed
        // tile of the same shape)
        direct_entry<256, 256, 16, 128, 64, 2, true, 1, true>(92),
        direct_entry<256, 128, 16, 64, 64, 2, true, 1, true>(91),
        direct_entry<128, 128, 16, 64, 64, 2, true, 1, true>(90),
        direct_entry<128, 128, 32, 64, 64, 2, true, 2, true>(89),   // 2 k-groups of 4 waves
        direct_entry<128, 64, 32, 64, 64, 2, true, 2, true>(88),    // 2 k-groups of 2 waves
        direct_entry<64, 128, 32, 64, 64, 2, true, 2, true>(88),    // 2 k-groups of 2 waves
    };
    *count = sizeof(tiles) / sizeof(tiles[0]);
    return tiles;
}

}  // namespace sg
