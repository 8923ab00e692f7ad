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
#define DIRECT_TILE(BM, BN, BK, WM, WN, NBUF, EDGES, KG, EFF) \
    direct_entry<BM, BN, BK, WM, WN, NBUF, EDGES, KG>(EFF),
#include "direct_tiles.inc"
#undef DIRECT_TILE
    };
    *count = sizeof(tiles) / sizeof(tiles[0]);
    return tiles;
}

}  // namespace sg
