// mfma_direct.hip -- the direct-load MFMA tiles for untransposed A: the tile
// table of the kernel templates in direct_kernel.hpp (B untransposed, and B
// transposed on the tiles compiled with edges).
#include "direct_kernel.hpp"

namespace sg {

bool direct_applies(const Problem &p, int bm, int bn, int bk, bool edges) {
    const long long a_rows = p.trans_a ? bk : bm;   // rows of A a tile's panel spans
    const long long b_rows = p.trans_b ? bn : bk;   // ... of B
    const bool offsets_fit =
        a_rows * p.lda * 4 < (1LL << 31) && b_rows * p.ldb * 4 < (1LL << 31);
    if (edges) return offsets_fit;
    return offsets_fit && p.M % bm == 0 && p.N % bn == 0 && p.K % bk == 0 && p.K >= bk;
}

const TileEntry *mfma_direct_tiles(int *count) {
    static const TileEntry tiles[] = {
        // argument: % of the fp32 peak measured at 4096^3
        direct_entry<256, 256, 16, 64, 128, 2, false>(93),
        direct_entry<256, 256, 16, 128, 64, 2, true>(92),
        direct_entry<256, 128, 16, 64, 64, 2, true>(91),
        direct_entry<128, 128, 16, 32, 64, 2, true>(92),
        direct_entry<128, 128, 16, 64, 64, 2, true>(90),
        direct_entry<256, 256, 32, 64, 128, 2, false>(93),
        direct_entry<256, 256, 32, 128, 64, 2, false>(93),
        direct_entry<128, 128, 32, 32, 64, 2, false>(91),
        direct_entry<64, 64, 32, 32, 64, 2, true, 2>(90),     // 2 k-groups of 2 waves
        direct_entry<128, 64, 32, 32, 64, 2, true, 2>(90),    // 2 k-groups of 4 waves
        direct_entry<64, 128, 32, 32, 64, 2, true, 2>(91),    // 2 k-groups of 4 waves
        direct_entry<128, 128, 32, 64, 64, 2, true, 2>(89),   // 2 k-groups of 4 waves
    };
    *count = sizeof(tiles) / sizeof(tiles[0]);
    return tiles;
}

}  // namespace sg
